"""Pins of the byte accountant (synth/accounting.py), which every reported
bandwidth and "% of peak" divides by.

Two independent anchors:
* parameter counts and sizes the pages print for the drafter
  (alphaneural.io "kimi-k3-dspark-gguf": 2.4B parameters, 4.45 GB without the
  embedding and 1.17B embedding parameters; huggingface.co
  "Kimi-K3-DSpark-NVFP4", "What is quantized to what": 3.56 B parameters in
  all, of which the quantised set is 2.19 B, 61 %);
* the per-workload byte totals worked out by hand from the tensor shapes
  (34 bytes per Q8_0 block of 32, FP8 one byte per weight plus an fp32 scale
  per row, bf16 2 bytes, fp32 4 bytes; every weight and cache row once).
"""
import numpy as np
import pytest

from synth import accounting as A, configs as C


def _params(m, names):
    return sum(int(np.prod(C.tensor_shape(m, n))) for n in names)


def test_parameter_counts_match_printed_sizes():
    m = C.FULL
    names = C.tensor_names(m)
    body = [n for n in names if n != "lm_head"]
    total = _params(m, body)
    # the confidence head here reads the hidden state and the Markov feature
    # (7168 + 256 weights + 1 bias); a plain 7168 + 1 head gives the printed sum
    plain = total - m.markov_rank
    assert plain == 2_387_907_585
    assert round(plain / 1e9, 1) == 2.4                       # "2.4B params"
    assert round(2 * plain / 2**30, 2) == 4.45                # "(4.45 GB)" in bf16, GiB
    embed = m.vocab * m.hidden
    assert embed == 1_174_405_120                              # "1.17B" embedding
    assert round((plain + embed) / 1e9, 2) == 3.56             # "3.56 B"
    quant = [n for n in names if n.split(".")[-1] in ("fc", "q_b", "o", "gate", "up", "down")]
    qp = _params(m, quant)
    assert qp == 2_186_280_960
    assert round(qp / 1e9, 2) == 2.19 and round(100 * qp / (plain + embed)) == 61


@pytest.mark.parametrize("wl,want", [
    (C.CFG1, 21_628_164),   # itemised in test_cfg1_items_by_hand
    (C.CFG2, 207_099_904),
    (C.CFG3, 5_039_000_068),
    (C.CFG4, 7_607_683_588),
])
def test_pass_bytes_by_hand(wl, want):
    assert A.total_bytes(wl) == want


def test_cfg1_items_by_hand():
    # hidden 512, 1 layer, 8 heads, q_lora 128, latent 64 + 16, nope 32, v 32,
    # inter 1024, vocab 4096, Markov rank 16, ctx 256, everything fp32
    params = {
        "fc": 512 * 5 * 512, "fc_norm": 512, "L0.in_norm": 512, "L0.q_a": 128 * 512, "L0.q_a_norm": 128,
        "L0.kv_a": 80 * 512, "L0.kv_a_norm": 64, "L0.q_b": 8 * 48 * 128, "L0.kv_b": 8 * 64 * 64,
        "L0.o": 512 * 8 * 32, "L0.post_norm": 512, "L0.gate": 1024 * 512, "L0.up": 1024 * 512,
        "L0.down": 512 * 1024, "final_norm": 512, "lm_head": 4096 * 512, "markov_w1": 7 * 16,
        "markov_w2": 4096 * 16, "conf_w": 512 + 16, "conf_b": 1, "kv_cache": 256 * 80, "captured": 5 * 7 * 512,
    }
    pb = A.pass_bytes(C.CFG1)
    assert pb == {k: 4 * v for k, v in params.items()}
    assert sum(pb.values()) == 21_628_164


def test_cfg3_items_by_hand():
    pb = A.pass_bytes(C.CFG3)
    H, L = 7168, 5
    q8 = lambda r, c: r * c // 32 * 34
    assert pb["fc"] == q8(H, 5 * H) == 272_957_440
    assert sum(pb[f"L{l}.q_a"] + pb[f"L{l}.kv_a"] for l in range(L)) == 151_388_160
    assert sum(pb[f"L{l}.q_b"] for l in range(L)) == 100_270_080
    assert sum(pb[f"L{l}.kv_b"] for l in range(L)) == 83_886_080
    assert sum(pb[f"L{l}.o"] for l in range(L)) == 311_951_360
    assert sum(pb[f"L{l}.gate"] + pb[f"L{l}.up"] for l in range(L)) == 1_091_829_760
    assert sum(pb[f"L{l}.down"] for l in range(L)) == 545_914_880
    assert pb["lm_head"] == 2_348_810_240
    assert pb["markov_w2"] == 83_886_080
    assert pb["markov_w1"] == 7 * 256 * 2                      # gathered rows only
    assert pb["kv_cache"] == 5 * 8192 * 576 * 2 == 47_185_920
    assert pb["captured"] == 5 * 7 * H * 2 == 501_760


def test_cfg5_bytes_by_hand():
    wl = C.CFG5
    m = wl.model
    fp8 = lambda r, c: r * c + 4 * r
    want = fp8(m.hidden, 5 * m.hidden) + 5 * (fp8(m.n_heads * 192, m.q_lora) + fp8(m.hidden, 8192)
                                              + 2 * fp8(m.inter, m.hidden) + fp8(m.hidden, m.inter))
    want += 5 * 2 * (m.q_lora + m.latent) * m.hidden + 5 * 2 * 64 * 256 * 512
    want += 2 * m.vocab * m.hidden + 2 * m.vocab * 256 + 2 * 16 * 7 * 256
    want += 4 * (2 * m.hidden + 5 * (2 * m.hidden + m.q_lora + m.kv_lora) + m.hidden + 256 + 1)
    want += 5 * wl.total_ctx * 576 * 2 + 16 * 5 * 7 * m.hidden * 2
    assert A.total_bytes(wl) == want


def test_lm_head_launch_bytes():
    # weights once, the fp32 normed hidden rows in, the fp32 logits out
    assert A.lm_head_launch_bytes(C.CFG3) == 2 * 163840 * 7168 + 4 * 7 * 7168 + 4 * 7 * 163840
