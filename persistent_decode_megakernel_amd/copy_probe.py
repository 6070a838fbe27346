"""Plain device-to-device copy of a known size, for calibrating HBM byte counters.

Run under `rocprofv3 --pmc FETCH_SIZE` (then WRITE_SIZE): the counters of this
copy, compared with its exact byte count, give the scale applied to the
engine kernel's counter readings.
"""
import sys

import torch

NBYTES = 1 << 30  # 1 GiB read and 1 GiB written per copy


def main():
    n = int(sys.argv[1]) if len(sys.argv) > 1 else NBYTES
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(f"copied {n} bytes x 3")


if __name__ == "__main__":
    main()
