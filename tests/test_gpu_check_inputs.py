"""GPU tests of gqa_decode_check_inputs: the device-side check of the decode calls'
device-resident preconditions (lengths in [q_len, capacity]; block-table entries that
a step reads in [0, num_pages)). Every case is a valid call of the check itself: the
planted mistakes are in the data it inspects, which no decode kernel is given here."""
import numpy as np
import pytest

torch = pytest.importorskip("torch")

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import gqa_kv_cache_03_amd  # noqa: F401  (fails loudly if the library is missing)


def dev(a):
    return torch.as_tensor(np.asarray(a, dtype=np.int32), device="cuda")


CLEAN = {"bad_lengths": 0, "bad_entries": 0, "first_bad_sequence": None, "first_bad_entry": None}


def test_valid_contiguous_inputs_report_nothing():
    from gqa_kv_cache_03_amd import check_inputs
    r = check_inputs(dev([4, 100, 4096]), q_len=4, capacity=4096)
    assert r == CLEAN


def test_bad_lengths_are_counted_and_the_first_named():
    from gqa_kv_cache_03_amd import check_inputs
    # q_len 4, capacity 512: 3 < q_len, 0, 513 > capacity; 4 and 512 are the edges and fine
    r = check_inputs(dev([4, 3, 512, 0, 513, 7]), q_len=4, capacity=512)
    assert r == {"bad_lengths": 3, "bad_entries": 0, "first_bad_sequence": 1, "first_bad_entry": None}


def test_valid_paged_inputs_report_nothing():
    from gqa_kv_cache_03_amd import check_inputs
    P, mb = 16, 8
    table = np.full((3, mb), -1, dtype=np.int32)   # entries past ceil(L/P) are never read
    table[0, :1] = [5]                              # L = 1
    table[1, :8] = np.arange(8)                     # L = 128: every entry
    table[2, :3] = [9, 10, 11]                      # L = 33
    r = check_inputs(dev([1, 128, 33]), dev(table), q_len=1, page_size=P, num_pages=12)
    assert r == CLEAN


def test_bad_table_entries_among_those_read():
    from gqa_kv_cache_03_amd import check_inputs
    P, mb, pages = 32, 6, 20
    lens = [70, 200, 33, 5]                         # ceil(L/P) = 3, 7 -> clamped to capacity 192: 6, 2, 1
    table = np.zeros((4, mb), dtype=np.int32)
    table[0, :3] = [1, 2, 3]
    table[0, 3:] = [-7, 99, 1000]                   # past the read range: not counted
    table[1, :] = [4, 5, -1, 6, 20, 7]              # -1 at k=2, 20 = num_pages at k=4
    table[2, :2] = [8, 9]
    table[3, 0] = -2                                # the one entry L = 5 reads
    r = check_inputs(dev(lens), dev(table), q_len=1, page_size=P, num_pages=pages)
    assert r["bad_lengths"] == 1 and r["first_bad_sequence"] == 1   # 200 > capacity 192
    assert r["bad_entries"] == 3
    assert r["first_bad_entry"] == 1 * mb + 2


def test_the_report_is_cleared_by_every_call():
    from gqa_kv_cache_03_amd import check_inputs
    bad = check_inputs(dev([0, 0]), q_len=1, capacity=64)
    assert bad["bad_lengths"] == 2
    assert check_inputs(dev([1, 64]), q_len=1, capacity=64) == CLEAN


def test_a_full_size_workload_passes_its_own_check():
    from gqa_kv_cache_03_amd import check_inputs
    from gqa_synth import WORKLOADS
    from gqa_synth.generate import draw_block_table, draw_lengths
    wl = WORKLOADS["paged16_bf16_B64_H32_G4_d128_n8k_64k"]
    lens = draw_lengths(wl)
    table, num_pages = draw_block_table(wl, lens)
    r = check_inputs(dev(lens), dev(table), q_len=wl.q_len, page_size=wl.page_size, num_pages=num_pages)
    assert r == CLEAN
