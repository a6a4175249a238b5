"""Precision budget of the 4-bit kernels' f16 codebook, on the CPU with the fp64 oracle.

The 4-bit kernels contract q with K in f16: the 16 centroids are rounded to f16 in the
table (11 significant bits).  On a long-context batch with the x20 outlier query channels
(the recipe of the long-context workload), the oracle run with f16-rounded centroids stays
within 3e-3 of the exact one, which leaves the rest of the 1e-2 bound to the bf16 rounding
of out (about 8e-3 where |out| reaches 2-4).  bf16-rounded centroids (8 bits) would use the
whole bound by themselves, which is why the table is f16."""

import numpy as np
import torch

import oracle
import workloads


def test_f16_codebook_error_budget():
    lens = (16384, 24000)
    wl = workloads.small_workload(name="budget", num_seqs=2, num_kv_heads=4, query_group_size=16,
                                  kv_block_size=32, seq_lens=lens, seed=0x5EED0005,
                                  outlier_frac=0.01)
    inp = workloads.make_inputs_tq4(wl, device="cpu", seq_lens=lens)

    def run(centroids):
        return oracle.decode_tq4(inp.q, inp.cache, centroids, inp.block_tables, inp.seq_lens,
                                 inp.softmax_scale, 4, 32, nthreads=8)

    exact = run(inp.centroids)
    err_f16 = np.abs(run(inp.centroids.to(torch.float16).float()) - exact).max()
    err_bf16 = np.abs(run(inp.centroids.to(torch.bfloat16).float()) - exact).max()
    assert np.abs(exact).max() > 1.0  # the outliers make |out| large, as on the workload
    assert err_f16 <= 3e-3, err_f16
    assert err_bf16 >= 4 * err_f16, (err_bf16, err_f16)
