"""The benchmark's algorithmic byte and operation counts (the numerators of its roofline
figures), checked against counts written out by hand for the OLMoE- and GLM-scale shapes."""
import bench
import synth


def _wl(i, **kw):
    w = dict(synth.WORKLOADS[i])
    w.update(kw)
    return w


def test_expert_gateup_bytes_per_format():
    # one OLMoE-scale expert (H = 2048, F = 1024): 2F rows of H inputs plus their scales
    H, F = 2048, 1024
    per_row = {  # packed bytes + scale bytes of one gate/up row
        (4, 0): H // 2 + 4,            # int4, one fp32 scale per row
        (4, 64): H // 2 + 4 * H // 64, # int4, one fp32 scale per 64 inputs
        (8, 0): H + 4,
        (2, 0): H // 4 + 4,
        (40, 32): H // 2 + H // 32,    # MXFP4: 4-bit codes, one E8M0 byte per 32 inputs
    }
    for (wb, sg), row in per_row.items():
        wl = _wl(1, wbits=wb, scale_group=sg)
        # U = 1 expert, no tokens: only the weights
        got = bench.gateup_bytes(wl, 1, 0, pairs=0)
        assert got == 2 * F * row, (wb, sg, got)
    assert bench.gateup_bytes(_wl(1), 1, 0, pairs=0) == 2_105_344  # 2.11 MB per expert


def test_gateup_bytes_add_activations_and_h():
    wl = _wl(1)  # OLMoE decode, no shared expert
    T, pairs, U = 16, 128, 55
    w = U * 2 * 1024 * (1024 + 4)
    acts = T * (2048 + 4 * 2048 // 32)          # Q8_0 codes + one fp32 scale per 32
    h = pairs * (1024 + 4 * 1024 // 32)         # hq + hd of every pair
    assert bench.gateup_bytes(wl, U, T, pairs) == w + acts + h


def test_layer_weight_bytes_glm_shared():
    wl = _wl(2)  # GLM decode: H = 6144, F = 2048, shared expert
    U = 10
    per = 2 * 2048 * (3072 + 4) + 6144 * (1024 + 4)
    assert bench.layer_weight_bytes(wl, U) == (U + 1) * per


def test_gateup_ops_counts_pairs_and_shared_rows():
    wl = _wl(3)  # GLM prefill: shared expert
    T = 2048
    assert bench.gateup_ops(wl, T) == 2 * (T * 8 + T) * 2 * 2048 * 6144
