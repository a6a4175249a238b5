"""Run every entry point of one build of oracle.c on small inputs (the library path is
argv[1]).  Used by test_sanitizers.py with a build under the address and undefined-behaviour
sanitizers, in a child process that preloads the sanitizer runtime."""

import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import oracle  # noqa: E402
import workloads  # noqa: E402


def main(lib_path: str) -> None:
    orc = oracle.Oracle(lib_path)
    for qg, bs, lens in ((8, 16, (1, 17, 300)), (6, 32, (0, 33, 257)), (16, 16, (5, 0, 64))):
        wl = workloads.small_workload(num_seqs=len(lens), num_kv_heads=2, query_group_size=qg,
                                      kv_block_size=bs, seq_lens=lens, seed=qg + bs)
        inp = workloads.make_inputs(wl, device="cpu", seq_lens=lens)
        args = (inp.q, inp.k_cache, inp.v_cache, inp.kv_scales, inp.block_tables, inp.seq_lens,
                inp.softmax_scale)
        full = orc.decode(*args, nthreads=3)
        units = orc.decode(*args, units=[(2, 1), (0, 0)])
        assert np.array_equal(units[0], full[2, qg:2 * qg])
        o, m, l = orc.partials(*args, num_partitions=2, partition_tokens=256)
        merged = orc.merge(o, m, l, inp.seq_lens, 256)
        assert np.allclose(merged, full, rtol=1e-12, atol=1e-12)
        t4 = workloads.make_inputs_tq4(wl, device="cpu", seq_lens=lens)
        out4 = orc.decode_tq4(t4.q, t4.cache, t4.centroids, t4.block_tables, t4.seq_lens,
                              t4.softmax_scale, 2, bs, nthreads=2)
        assert np.all(np.isfinite(out4))
        orc.dequant_tq4(t4.cache, t4.centroids, 2, 128, bs, 0, 1, bs - 1)
    codes = np.arange(256, dtype=np.uint8)
    vals = orc.dec_e4m3fn(codes)
    finite = np.isfinite(vals)
    assert np.array_equal(orc.enc_e4m3fn(vals[finite].astype(np.float32)), codes[finite])
    orc.dec_bf16(np.arange(0, 65536, 257, dtype=np.uint16))
    orc.dec_f16(np.arange(0, 65536, 257, dtype=np.uint16))
    rng = np.random.default_rng(3)
    T, Hkv, BS, NB = 7, 3, 16, 4
    kn = rng.integers(0, 65536, size=(T, Hkv, 128), dtype=np.uint16) & 0xBFFF  # finite bf16
    vn = rng.integers(0, 65536, size=(T, Hkv, 128), dtype=np.uint16) & 0xBFFF
    slots = np.array([0, 5, -1, 63, 17, 2, 40], dtype=np.int32)
    kc = np.zeros((NB, Hkv, BS, 128), dtype=np.uint8)
    sc = np.zeros((NB, Hkv, 2, BS), dtype=np.float32)
    orc.kv_write(kn, vn, slots, kc, kc.copy(), sc)
    print("oracle_calls: done", flush=True)


if __name__ == "__main__":
    main(sys.argv[1])
