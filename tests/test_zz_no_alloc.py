"""sparse_mla_decode_noalloc: the decode step with its split partials in the
library's own device scratch (no allocation by the library or the caller beyond
inputs and outputs).  Its outputs must equal sparse_mla_decode's, given caller
partial buffers, on the same inputs: bit for bit, since the same kernels run on the
same values.  Two calls in a row, the second smaller, so stale partials of the first
call sit in the scratch during the second.  A shape whose partials exceed the
scratch is rejected before anything runs."""
import numpy as np
import pytest

from sparse_mla_decode_top_amd import workloads as W
from tests import _harness as H

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu


def _both(dev, S, out_kind):
    """(sparse_mla_decode with caller buffers, sparse_mla_decode_noalloc) outputs."""
    import sparse_mla_decode_top_amd as smla
    inp = dev.inp
    s_q, h_q = inp.s_q, inp.h_q
    res = []
    for noalloc in (False, True):
        if out_kind == "fp8":
            out = torch.full((s_q, h_q, 512), 0x7F, device="cuda", dtype=torch.uint8)
            scale = torch.full((s_q,), float("nan"), device="cuda")
        else:
            out = torch.full((s_q, h_q, 512), float("nan"), device="cuda",
                             dtype=torch.float32 if out_kind == "f32" else torch.bfloat16)
            scale = None
        lse = torch.full((s_q, h_q), float("nan"), device="cuda")
        if noalloc:
            smla.sparse_mla_decode_noalloc(dev.q, dev.kv, dev.indices, S, inp.scale, out, kv_scale=dev.kv_scale,
                                           sink=dev.sink, out_scale=scale, lse_out=lse)
        else:
            o_acc = lse_acc = None
            if S > 1:
                o_acc = torch.empty((S, s_q, h_q, 512), device="cuda")
                lse_acc = torch.empty((S, s_q, h_q), device="cuda")
            smla.sparse_mla_decode(dev.q, dev.kv, dev.indices, S, inp.scale, kv_scale=dev.kv_scale, sink=dev.sink,
                                   o_accum=o_acc, lse_accum=lse_acc, out=out, out_scale=scale, lse_out=lse)
        torch.cuda.synchronize()
        r = {"out": out.view(torch.uint8 if out_kind == "fp8" else out.dtype).cpu(), "lse": lse.cpu().numpy()}
        if scale is not None:
            r["scale"] = scale.cpu().numpy()
        res.append(r)
    return res


@pytest.mark.parametrize("first,second", [(("small16", 4, "bf16"), ("single", 10, "f32")),
                                          (("fp8_16", 8, "fp8"), ("fp8_1", 8, "fp8"))])
def test_noalloc_equals_sparse_mla_decode_on_two_calls(first, second):
    for name, S, kind in (first, second):
        print(f"[case] noalloc {name} S={S} out={kind}", flush=True)
        dev = H.DeviceInputs(H.inputs_for(name, 0))
        ref, got = _both(dev, S, kind)
        assert torch.equal(ref["out"], got["out"])
        assert np.array_equal(ref["lse"], got["lse"])
        if kind == "fp8":
            assert np.array_equal(ref["scale"], got["scale"])
        if kind == "f32":
            O_ref, L_ref = H.oracle_direct(name, 0)
            H.assert_o_close(got["out"].numpy().astype(np.float64), H.oracle_final(dev.inp, O_ref, L_ref))
            H.assert_lse_close(got["lse"], L_ref)


def test_noalloc_direct_path_and_scratch_limit():
    import sparse_mla_decode_top_amd as smla
    from sparse_mla_decode_top_amd import binding as B
    print("[case] noalloc direct and limit", flush=True)
    dev = H.DeviceInputs(H.inputs_for("small6", 0))
    ref, got = _both(dev, 1, "bf16")                 # num_splits = 1: the direct path, no scratch
    assert torch.equal(ref["out"], got["out"]) and np.array_equal(ref["lse"], got["lse"])
    # 6 tokens x 64 heads x 64 splits of partials: 50 MB > 32 MiB of scratch
    inp = dev.inp
    need = smla.smla_partial_bytes(inp.s_q, inp.h_q, 64)
    assert need > B.NOALLOC_SCRATCH_BYTES
    out = torch.full((inp.s_q, 64, 512), float("nan"), device="cuda")
    with pytest.raises(smla.SmlaError) as e:
        smla.sparse_mla_decode_noalloc(dev.q, dev.kv, dev.indices, 64, inp.scale, out, sink=dev.sink)
    assert e.value.status == 6
    torch.cuda.synchronize()
    assert torch.isnan(out).all()                    # nothing ran
