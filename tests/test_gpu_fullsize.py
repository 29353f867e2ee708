"""GPU parity at the full workload sizes, in the launch configuration the benchmark
times (the library's default plan, one call over the whole batch).

Every output element is compared with the fp64 oracle: the oracle computes each
(sequence, KV group) unit on its own, from exactly the cache rows that unit reads,
on host threads, and each unit's output slice must pass the graded tolerance and the
relative-L2 gate. NaN fills every cache slot the step must not read, so a stray read
shows up as a non-finite output.
"""
import pytest

torch = pytest.importorskip("torch")

from gpu_cases import all_units_parity  # noqa: E402
from gqa_synth import WORKLOADS, make_inputs  # noqa: E402

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gqa_kv_cache_03_amd  # noqa: F401  (fails loudly if the library is missing)


def _log(msg):
    print(msg, flush=True)


@pytest.mark.parametrize("name", [n for n, w in WORKLOADS.items() if not w.d_c])
def test_full_size_parity_every_unit(name):
    from gqa_kv_cache_03_amd import gqa_decode, plan
    wl = WORKLOADS[name]
    _log(f"[fullsize] {name}: generating")
    inp = make_inputs(wl, device="cuda")
    pl = plan(inp.q, inp.k_cache, inp.block_table, causal=wl.causal)
    _log(f"[fullsize] {name}: decode, plan {pl['policy']} / {pl['schedule']} / {pl['workgroups']} workgroups")
    out = gqa_decode(inp.q, inp.k_cache, inp.v_cache, inp.seq_lens, inp.block_table,
                     scale=wl.scale, causal=wl.causal)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(out).all()), f"{name}: non-finite output"
    worst = all_units_parity(inp, out, name, log=_log)
    assert worst["units"] == wl.B * wl.G
    del inp, out
    torch.cuda.empty_cache()


@pytest.mark.parametrize("name", ["llama3_8b_decode_bf16_B16_H32_G8_d128_n4096",
                                  "paged16_bf16_B64_H32_G4_d128_n8k_64k",
                                  "causal4_bf16_B8_H32_G1_d128_n131072p4"])
def test_full_size_append_every_unit(name):
    """The fused append at full size, default plan: the new tokens' K/V come from k_new /
    v_new (their cache slots hold NaN on entry). Afterwards the cache equals the generated
    one bit for bit, and every (sequence, group) unit of the output matches the oracle
    over it."""
    from gqa_kv_cache_03_amd import gqa_decode_append
    from test_gpu_append import split_new_rows
    wl = WORKLOADS[name]
    _log(f"[fullsize append] {name}: generating")
    inp = make_inputs(wl, device="cuda")
    full_k, full_v = inp.k_cache.clone(), inp.v_cache.clone()
    k_new, v_new = split_new_rows(inp)
    out = gqa_decode_append(inp.q, k_new, v_new, inp.k_cache, inp.v_cache, inp.seq_lens, inp.block_table,
                            scale=wl.scale, causal=wl.causal)
    torch.cuda.synchronize()
    assert torch.equal(inp.k_cache.view(torch.int16), full_k.view(torch.int16)), "K cache bytes"
    assert torch.equal(inp.v_cache.view(torch.int16), full_v.view(torch.int16)), "V cache bytes"
    del full_k, full_v
    worst = all_units_parity(inp, out, name + " +append", log=_log)
    assert worst["units"] == wl.B * wl.G
    del inp, out
    torch.cuda.empty_cache()
