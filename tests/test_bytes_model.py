"""The bytes model against the numbers the pages print.

tuna-fish README, "Inference estimation": the decode bytes formula and its
inputs; "Inference speedtest": it/s and GB/s pairs (the page's GB is 2^30
bytes, at 2 bytes per element for bf16 and 1 for fp8) and prefill tok/s with
seconds; "training estimation": the fast AR parameter count. Our own
parameter enumeration (the canonical tensor list) must reproduce the pages'
fast AR counts exactly, once with a 4096-entry head and once with 1024 entries.
"""
import json
import os

import pytest

from dar_decode_frame_amd import bytes_model as bm
from synth import DIMS, tensor_specs

GOLD = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "pages_numbers.json")))


def test_pages_formula_reproduces_printed_total():
    e = GOLD["inference_estimation"]
    n = bm.pages_decode_elements(e["slow_params_wo_emb"], e["fast_params_wo_emb"], e["n_layers_slow"],
                                 e["n_layers_fast"], e["c_kv"], e["max_length"], e["fast_kv_len"],
                                 e["fast_passes"], e["batch"])
    assert n == e["decode_elements"]
    assert round(n * 2 / bm.GIB, 2) == e["bf16_gib_printed"]


@pytest.mark.parametrize("pt", GOLD["speedtest"]["decode_points"], ids=lambda p: f"{p['gpu']}-{p['it_s']}")
def test_printed_gb_s_is_it_s_times_step_bytes_in_gib(pt):
    e = GOLD["inference_estimation"]
    per_it = e["decode_elements"] * GOLD["speedtest"]["bytes_per_element"][pt["q"]] / bm.GIB
    # the printed it/s carries one decimal: the implied it/s must round to it
    implied = pt["gb_s"] / per_it
    assert abs(implied - pt["it_s"]) <= 0.05 + 1e-9


@pytest.mark.parametrize("pt", GOLD["speedtest"]["prefill_points"], ids=lambda p: f"{p['gpu']}-{p['tok_s']}")
def test_printed_prefill_seconds(pt):
    assert round(pt["tokens"] / pt["tok_s"], 3) == pytest.approx(pt["seconds"], abs=1e-9)


def test_fast_param_enumeration_matches_pages():
    dual = DIMS["s2pro_dual"]
    assert bm.fast_params_wo_emb(dual) == GOLD["training_estimation"]["fast_params_wo_emb"]
    assert bm.fast_params_wo_emb(dual, fast_head_rows=1024) == GOLD["inference_estimation"]["fast_params_wo_emb"]
    # the same count straight from the canonical tensor list
    n = sum(int(__import__("numpy").prod(s)) for name, s, k in tensor_specs(dual) if name.startswith("fast.") and k != "emb")
    assert n == GOLD["training_estimation"]["fast_params_wo_emb"]


def test_slow_param_count_near_pages():
    # ours: 36 blocks + final norm + the 4096 x 2560 codebook-0 head; the page's
    # slow count is larger by 11,776 = 36*2*128 + 2560 (tensors the pages never
    # name; 3.2e-6 relative)
    c = bm.param_counts(DIMS["s2pro_dual"])
    ours = c["slow_layers"] + c["slow_final_norm"] + c["slow_head"]
    assert ours == 3_643_988_480
    assert GOLD["inference_estimation"]["slow_params_wo_emb"] - ours == 11_776


def test_frame_bytes_full_shape():
    dual, slow = DIMS["s2pro_dual"], DIMS["s2pro_slow"]
    assert bm.kv_bytes_per_position(dual) == 147_456
    assert bm.frame_bytes(dual, "bf16", 1024) == 14_895_646_720
    assert bm.frame_bytes(dual, "bf16", 129) == 14_763_673_600
    assert bm.frame_bytes(dual, "fp8", 1024) == 7_543_638_016
    assert bm.slow_weight_bytes(dual, "fp8") == 3_659_084_800
    assert bm.fast_pass_bytes(dual, "fp8") == 414_741_504
    assert bm.frame_bytes(slow, "bf16", 0) == 7_287_976_960
    assert bm.fast_kv_bytes(dual) == 884_736
    # run sums match frame-by-frame sums
    assert bm.run_bytes(dual, "bf16", 129, 896) == sum(bm.frame_bytes(dual, "bf16", t) for t in range(129, 1025))


@pytest.mark.parametrize("name", ["s2pro_dual_cb16", "s2pro_dual_cb64"])
def test_continuous_workload_pool_covers_its_requests(name):
    """A continuous-batching workload's page pool holds every slot's longest
    request (prompt + frames + the slow step computed ahead), and no request
    passes the position limit of a paged slot (frames up to max_len - 2)."""
    import synth
    wl = synth.WORKLOADS[name]
    lens, frames, _ = synth.gen_requests(wl.requests, wl.prefill_len, wl.prefill_len_max, wl.frames_min,
                                         wl.decode_frames, wl.dims.vocab_c0, wl.prompt_seed, wl.length_seed)
    longest = int((lens + frames).max()) + 1
    assert longest <= wl.max_len - 1
    per_slot = -(-longest // wl.page_len)
    assert wl.batch * per_slot <= wl.n_pages - 1
    assert wl.max_len % wl.page_len == 0 and wl.max_len // wl.page_len <= 64
