"""Partition-size sweep of the fused decode step, to check the partition planner on a GPU.

For each batch of context lengths it builds a step of ``--layers`` layers (each layer its own
pages of one shared pool, as in a model; pool contents are random BF16 filled on the GPU), replays
the whole step from a HIP graph for every candidate partition size, and prints one JSON line per
batch: microseconds per layer for each size, the planner's choice, the best size and the ratio of
the planner's time to the best.  A final line summarises the ratios.

    python -m paged_kv_cache_pages_amd.plan_sweep [--layers 16] [--pps 4,6,8,...] [--seed 7]
"""

import argparse
import json

import numpy as np


def batches(rng):
    out = []
    for b in (1, 2, 4, 8, 16, 24):
        out.append((f"uniform 2048 x{b}", [2048] * b))
    for b in (4, 8, 16, 32):
        out.append((f"uniform 1024 x{b}", [1024] * b))
    for length in (256, 384, 512):
        for b in (1, 4, 16):
            out.append((f"uniform {length} x{b}", [length] * b))
    for b in (8, 17, 32, 64):
        out.append((f"geometric mean 256 x{b}", [int(min(2048, x)) for x in rng.geometric(1 / 256, b)]))
    for b in (8, 16, 32):
        out.append((f"uniform 1..2048 x{b}", [int(x) for x in rng.integers(1, 2049, b)]))
    return out


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--layers", type=int, default=16)
    ap.add_argument("--pps", default="4,6,8,10,12,16,20,24,32,48,64,128")
    ap.add_argument("--seed", type=int, default=7)
    ap.add_argument("--lengths", default="", help="extra batch: comma-separated context lengths")
    args = ap.parse_args()

    import torch

    import paged_kv_cache_pages_amd as pkv

    pps = [int(x) for x in args.pps.split(",")]
    rng = np.random.default_rng(args.seed)
    todo = batches(rng)
    if args.lengths:
        todo.append(("given lengths", [int(x) for x in args.lengths.split(",")]))
    cus = pkv.cu_count()
    ratios = []
    for name, lens in todo:
        lens = np.asarray(lens)
        batch, layers = len(lens), args.layers
        pages = (lens + 15) // 16
        total = int(pages.sum()) * layers
        perm = rng.permutation(total).astype(np.int32)
        tables = np.full((layers, batch, 128), -1, dtype=np.int32)
        k = 0
        for l in range(layers):
            for b in range(batch):
                tables[l, b, :pages[b]] = perm[k:k + pages[b]]
                k += pages[b]
        k_pool = torch.randn((total, 8, 16, 64), device="cuda").to(torch.bfloat16)
        v_pool = torch.randn((total, 8, 16, 64), device="cuda").to(torch.bfloat16)
        bt = [torch.from_numpy(tables[l]).cuda() for l in range(layers)]
        pos = torch.from_numpy((lens - 1).astype(np.int32)).cuda()
        q = [torch.randn((batch, 32, 64), device="cuda").to(torch.bfloat16) for _ in range(layers)]
        kn = [torch.randn((batch, 8, 64), device="cuda").to(torch.bfloat16) for _ in range(layers)]
        vn = [torch.randn((batch, 8, 64), device="cuda").to(torch.bfloat16) for _ in range(layers)]
        out = torch.empty((batch, 32, 64), dtype=torch.bfloat16, device="cuda")
        planned = pkv.plan_partition_pages(batch, 8, 128, num_cus=cus, max_context=int(lens.max()))
        res = {"batch": name, "B": batch, "max_context": int(lens.max()), "planned": planned}
        for pp in sorted(set(pps + [planned])):
            ws = torch.zeros(max(16, pkv.decode_workspace_bytes(batch, 32, 128, pp)), dtype=torch.uint8, device="cuda")

            def step():
                for l in range(layers):
                    pkv.decode_step(q[l], k_pool, v_pool, bt[l], pos, kn[l], vn[l], out, partition_pages=pp,
                                    workspace=ws)

            side = torch.cuda.Stream()
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):
                step()
            torch.cuda.current_stream().wait_stream(side)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for _ in range(4):
                    step()
            g.replay()
            torch.cuda.synchronize()
            ts = []
            for _ in range(5):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                g.replay()
                e1.record()
                torch.cuda.synchronize()
                ts.append(e0.elapsed_time(e1) / (4 * layers) * 1e3)
            res[str(pp)] = round(float(np.median(ts)), 2)
            del g
        best = min((p for p in res if p.isdigit()), key=lambda p: res[p])
        res["best"] = int(best)
        res["planned_vs_best"] = round(res[str(planned)] / res[best], 3)
        ratios.append(res["planned_vs_best"])
        print(json.dumps(res), flush=True)
        del k_pool, v_pool
        torch.cuda.empty_cache()
    print(json.dumps({"batches": len(ratios), "planned_vs_best_mean": round(float(np.mean(ratios)), 3),
                      "planned_vs_best_max": max(ratios), "layers": args.layers, "cus": cus}), flush=True)


if __name__ == "__main__":
    main()
