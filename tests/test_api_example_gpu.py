"""The decode loop of the README, at a small size, through the public binding
only: an engine, the history appended, then steps with their appends and the
gathers of every layer; every gathered byte must equal the rows appended for the
selected addresses, and the statistics must add up."""

import numpy as np
import pytest

pytestmark = pytest.mark.gpu


def test_readme_decode_loop():
    import torch
    from serving_pb_lru_amd import Engine

    torch.cuda.set_device(0)
    rng = np.random.default_rng(7)
    layers, row_bytes, n_sets, k, steps = 3, 656, 2, 64, 6
    hist = 1500
    N, P = hist + steps * n_sets, 600
    rows_of = {}

    def rows_for(las):
        out = np.empty((len(las), layers, row_bytes), np.uint8)
        for i, la in enumerate(las):
            if la not in rows_of:
                rows_of[la] = rng.integers(0, 256, (layers, row_bytes), dtype=np.uint8)
            out[i] = rows_of[la]
        return out

    eng = Engine(num_groups=1, layers=layers, row_bytes=row_bytes, ring=8, logical_capacity=N,
                 gpu_slots=P, host_slots=N - P, max_sets=n_sets, max_k=k)
    try:
        history = np.arange(hist, dtype=np.int32)
        eng.append(0, history, rows_for(history))
        alive = hist
        for step in range(steps):
            new = np.arange(alive, alive + n_sets, dtype=np.int32)
            alive += n_sets
            pick = np.stack([rng.choice(alive, size=k, replace=False) for _ in range(n_sets)]).astype(np.int32)
            pick[0, :3] = -1                                    # padding
            sel = torch.from_numpy(pick).cuda()
            eng.append_step(0, new, torch.from_numpy(rows_for(new)).cuda(), sel)
            kv0 = eng.gather(0, 0, sel)
            kv12 = eng.gather_layers(0, 1, 2, sel)
            stats = eng.sync()[0]
            flat = pick.reshape(-1)
            want = np.zeros((flat.size, layers, row_bytes), np.uint8)
            want[flat >= 0] = rows_for(flat[flat >= 0])
            assert np.array_equal(kv0.cpu().numpy().reshape(flat.size, row_bytes), want[:, 0])
            for l in (1, 2):
                assert np.array_equal(kv12[l - 1].cpu().numpy().reshape(flat.size, row_bytes), want[:, l])
            unique, hits, misses, _, _, invalid = stats
            assert invalid == 3 and hits + misses == unique == len(set(flat[flat >= 0].tolist()))
    finally:
        eng.close()
