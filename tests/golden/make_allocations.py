"""Write tests/golden/allocations.json: the oracle allocator's (r_T, r_F, b)
table for each workload and byte budget.

Calls only the seeded input generators and the oracle (spectra of each
grouped cache, then the single-multiplier allocator).  The timing benchmark and
the large-shape parity tests read this table to shape their synthetic caches.

    python tests/golden/make_allocations.py [config ...]     (default: 1 2)
"""
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from oracle import allocate as al  # noqa: E402
from oracle.compress import budget_for, cell_stats  # noqa: E402
from workloads import gen, get_config  # noqa: E402
from workloads.configs import mha7b_schedule  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "allocations.json")


def stats_for(cfg, seq):
    cells = []
    for g in range(cfg.n_groups):
        for tau in (0, 1):
            t0 = time.time()
            X = gen.kv_group(cfg, seq, g, tau)
            cells.append(cell_stats(X, cfg.factor_bytes))
            del X
            print(f"  cfg{cfg.idx} seq{seq} group{g} tau{tau}: spectra {time.time() - t0:.1f}s",
                  flush=True)
    return cells


def table(cfg, cells, ratio):
    budget = budget_for(ratio, cfg.n_layers, cfg.H, cfg.d, cfg.T)
    A = al.Allocator(cells)
    choice, lam = A.solve(budget)
    groups = [[list(choice[2 * g]), list(choice[2 * g + 1])] for g in range(cfg.n_groups)]
    nbytes = A.total_bytes(choice)
    return {"ratio": ratio, "budget": budget, "lambda": lam, "bytes": int(nbytes),
            "achieved_ratio": budget * ratio / nbytes, "surrogate": A.total_surrogate(choice),
            "groups": groups}


def main(keys):
    data = json.load(open(OUT)) if os.path.exists(OUT) else {}
    for k in keys:
        cfg = get_config(k)
        entry = {"name": cfg.name, "tables": {}}
        if cfg.fixed is not None:
            entry["tables"]["fixed"] = {"groups": [[list(cfg.fixed), list(cfg.fixed)]] * cfg.n_groups}
        elif cfg.schedule == "mha-7b":
            entry["tables"]["fixed"] = {"groups": [[list(a), list(b)] for a, b in
                                                   (mha7b_schedule(g) for g in range(cfg.n_groups))]}
        else:
            seqs = range(cfg.batch) if cfg.batch > 1 else [0]
            for seq in seqs:
                cells = stats_for(cfg, seq)
                for r in cfg.budgets:
                    key = f"{r:g}x" + (f"/seq{seq}" if cfg.batch > 1 else "")
                    entry["tables"][key] = table(cfg, cells, r)
                    print(f"cfg{k} {key}: {entry['tables'][key]['groups']}", flush=True)
        data[str(k)] = entry
        with open(OUT, "w") as f:
            json.dump(data, f, indent=1)


if __name__ == "__main__":
    main([int(a) for a in sys.argv[1:]] or [0, 1, 2, 4])
