"""pa_decode_noalloc inside a captured HIP graph (the entry point is for
callers that cannot allocate, code under graph capture among them): a graph
holding one call is replayed several times, with the program's own eager
decode calls and synchronizations between the replays and the query changed
in place before the last one; every replay must give the bits of the eager
pa_decode on the inputs of that moment."""
import sys

import numpy as np
import pytest

from paged_kv_cache_349_amd import workloads as wl

pytestmark = pytest.mark.gpu


def _say(msg):
    print(msg, file=sys.stderr, flush=True)


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import paged_kv_cache_349_amd as pa
    pa.load_library()
    yield


# (config, sequences): 8 sequences are planned inside the attention kernel
# (two kernels per call); 128 sequences of the large batch take the planner
# launch (three kernels).
@pytest.mark.parametrize("cfg,num_seqs", [(3, None), (5, 128)])
def test_noalloc_decode_replays_in_a_graph(cfg, num_seqs):
    import torch
    import paged_kv_cache_349_amd as pa
    from paged_kv_cache_349_amd.device_io import upload
    w = wl.make_config(cfg, num_seqs=num_seqs)
    _say(f"graph capture: config {cfg}, {w.num_seqs} sequences")
    d = upload(w)
    pa.write_kv(d.k_cache, d.v_cache, d.k_new, d.v_new, d.slot_mapping)
    args = (d.q, d.k_cache, d.v_cache, d.block_tables, d.context_lens, float(w.scale),
            w.block_size)

    def eager():
        ref = torch.full_like(d.out, float("nan"))
        pa.decode(ref, *args)
        torch.cuda.synchronize()
        return ref

    out_g = torch.full_like(d.out, float("nan"))
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):          # first call outside the capture
        pa.decode_noalloc(out_g, *args)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=side):
        pa.decode_noalloc(out_g, *args)
    torch.cuda.synchronize()
    for rep in range(4):
        if rep == 3:
            d.q.neg_()                      # the graph reads the query of the moment
        expect = eager()
        out_g.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert pa.decode_check() == 0
        same = torch.equal(out_g.view(torch.int32), expect.view(torch.int32))
        _say(f"  replay {rep}: bitwise equal to the eager call: {same}")
        assert same
    del g
    torch.cuda.synchronize()
