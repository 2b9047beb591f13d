"""dt_build_noalloc (the entry point for callers that cannot allocate: its
scratch is the library's static per-device array) against dt_build, through
the C ABI: identical outputs, bit for bit, on two calls in a row, the second
with a smaller batch; and a configuration beyond the scratch is rejected
before anything is enqueued."""
import numpy as np
import pytest

import synthetic as S

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
if not torch.cuda.is_available():
    pytest.skip("no GPU", allow_module_level=True)

import conditional_draft_tree_amd as dtree  # noqa: E402

DEV = torch.device("cuda", 0)
KEYS = ("tokens", "parents", "depths", "scores", "mask", "count", "flags")


def _builder(cfg, B):
    # dt_build_noalloc runs the stepped expansion; dt_build of the same handle
    # is made to run it too, so the two are compared bit for bit
    return dtree.Builder(B, cfg["L"], cfg["V"], cfg["E"], cfg["H"], cfg["M"], cfg["n"], cfg["T"], cfg["dtype"],
                         1e-5, device=DEV, expand=dtree.DT_EXPAND_STEPPED)


def _noalloc(bld, t):
    out = bld._outputs()
    for v in out.values():  # garbage, so that nothing the call should write is left from before
        v.view(torch.uint8).fill_(0xA5)
    dtree.dt_build_noalloc(bld.handle, t["base"], t["emb"], t["w_ih"], t["w_hh"], t["b_ih"], t["b_hh"], t["C"],
                           t["h0"], out["tokens"], out["parents"], out["depths"], out["scores"], out["mask"],
                           out["count"], out["flags"])
    return out


def _np(out):
    return {k: (v.view(torch.int32) if v.dtype == torch.uint32 else v).cpu().numpy() for k, v in out.items()}


@pytest.mark.parametrize("name,variant", [("qwen3_4b_batched", "default"), ("qwen3_4b_batched", "strong")])
def test_noalloc_equals_build_on_two_calls_second_smaller(name, variant):
    cfg = S.CONFIGS[name]
    inp = S.make_inputs(cfg, seed=0, variant=variant)
    t = S.to_torch(inp, DEV)
    small_B = 9
    ts = dict(t)
    ts["base"] = t["base"][:small_B].contiguous()
    ts["h0"] = t["h0"][:small_B].contiguous() if t["h0"] is not None else None
    big, small = _builder(cfg, cfg["B"]), _builder(cfg, small_B)
    ref_big = _np(big.build(t["base"], t["emb"], t["w_ih"], t["w_hh"], t["b_ih"], t["b_hh"], t["C"], t["h0"]))
    ref_small = _np(small.build(ts["base"], ts["emb"], ts["w_ih"], ts["w_hh"], ts["b_ih"], ts["b_hh"], ts["C"],
                                ts["h0"]))
    got_big = _noalloc(big, t)      # first call: the whole batch
    got_small = _noalloc(small, ts)  # second call, same scratch: a smaller batch
    torch.cuda.synchronize()
    got_big, got_small = _np(got_big), _np(got_small)
    for k in KEYS:
        np.testing.assert_array_equal(got_big[k], ref_big[k], err_msg=f"B={cfg['B']}: {k}")
        np.testing.assert_array_equal(got_small[k], ref_small[k], err_msg=f"B={small_B}: {k}")
    print(f"noalloc {name}/{variant}: B={cfg['B']} then B={small_B} equal dt_build bit for bit", flush=True)
    big.close()
    small.close()


def test_noalloc_rejects_a_configuration_beyond_the_scratch():
    cfg = S.CONFIGS["stress"]  # B = 256, n = 64: more scratch than the static array holds
    bld = _builder(cfg, cfg["B"])
    out = bld._outputs()
    fake = torch.zeros(16, dtype=torch.uint8, device=DEV)  # never read: rejected before any launch
    with pytest.raises(ValueError, match="UNSUPPORTED.*scratch"):
        dtree.dt_build_noalloc(bld.handle, fake, fake, fake, fake, None, None, fake, None, out["tokens"],
                               out["parents"], out["depths"], out["scores"], out["mask"], out["count"], out["flags"])
    bld.close()
