"""qhead_q6k_static_scratch, the Q6_K entry point that allocates nothing
(its q8_1 activations live in a fixed per-GPU device array): its logits must
equal qhead_q6k's bit for bit (same kernels, same chunking), on two calls in a
row, the second smaller than the first, so that the second call finds the
first call's bytes in the array and must not depend on them."""

import numpy as np
import pytest

pytestmark = pytest.mark.gpu


def _case(seed, rows, hidden, vocab):
    import oracle
    import synth
    from gpu_helpers import dev_bf16, dev_u8

    wf = synth.weight_rows_f32(synth.NVFP4_Q6K_129280X7168, seed, seed + vocab,
                               vocab=seed + vocab, hidden=hidden)
    blocks = oracle.prep_q6k_rows(wf)
    x = synth.activations_bf16(synth.NVFP4_Q6K_129280X7168, rows, hidden=hidden, max_rows=rows)
    return dev_u8(blocks), dev_bf16(x), blocks, x


def test_static_scratch_matches_workspace_entry_point():
    import oracle
    import torch
    from gpu_helpers import assert_within_bound, host_bits, log

    import quantized_weight_decode_amd as qh

    # first call: 11 rows (chunks 8 + 3), hidden 1280; second: 3 rows, hidden 512
    for seed, rows, hidden, vocab in ((0, 11, 1280, 1001), (5000, 3, 512, 300)):
        log(f"static-scratch Q6_K: rows {rows} hidden {hidden} vocab {vocab}")
        bd, xd, blocks, x = _case(seed, rows, hidden, vocab)
        got = host_bits(qh.q6k_static_scratch(bd, xd))
        ref_bits = host_bits(qh.q6k(bd, xd))
        torch.cuda.synchronize()
        assert np.array_equal(got, ref_bits), f"rows {rows}: differs from qhead_q6k"
        ref, ad = oracle.q6k_ref(blocks, oracle.quant_q8_1(x), hidden)
        assert_within_bound(got, ref, ad, f"static-scratch Q6_K rows {rows}")
