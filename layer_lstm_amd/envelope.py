"""The shapes the kernels take on the current device, as a short text table
for profiles/.

    python -m layer_lstm_amd.envelope [--out FILE]

For fp32 and bf16 storage (fp16 takes the bf16 layouts) and a range of
hidden sizes, the batch sizes among powers of two for which lstm_query
finds a layout of the persistent recurrences (T = 16, I = 256; T and I
change only the T*B and I bounds stated in include/lstm.h).  No kernel
runs.
"""
from __future__ import annotations

import argparse
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HS = (64, 128, 256, 384, 512, 640, 768, 896, 1024, 1280, 1536, 1792, 2048)
BS = (1, 2, 4, 8, 16, 32, 64, 128, 256, 512, 1024, 2048, 4096, 8192)


def main(argv=None):
    from layer_lstm_amd import lstm
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--out", default=None)
    args = ap.parse_args(argv)
    out_rel = os.path.relpath(os.path.abspath(args.out), ROOT) if args.out else None
    lines = ["Shapes the kernels take (lstm_query finds a layout), one MI355X", "",
             "command: python -m layer_lstm_amd.envelope" + (f" --out {out_rel}" if out_rel else ""), "",
             "largest batch B (powers of two up to 8192) per hidden size H; T = 16, I = 256", "",
             f"{'H':>6s} {'fp32':>8s} {'bf16/fp16':>10s}"]
    for H in HS:
        row = []
        for code in (lstm.F32, lstm.BF16):
            best = 0
            for B in BS:
                try:
                    lstm.query(lstm.make_shape(16, B, 256, H, code))
                    best = B
                except lstm.LstmError:
                    pass
            row.append(str(best) if best else "-")
        lines.append(f"{H:6d} {row[0]:>8s} {row[1]:>10s}")
    text = "\n".join(lines) + "\n"
    if args.out:
        with open(args.out, "w") as f:
            f.write(text)
    print(text, flush=True)


if __name__ == "__main__":
    main()
