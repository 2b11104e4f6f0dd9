"""Plain device-to-device copy of a known size, used to scale the FETCH_SIZE and
WRITE_SIZE hardware counters into bytes (three 1 GiB copies)."""

import torch

if __name__ == "__main__":
    a = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    a.fill_(1)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print("copied 3 x 1 GiB device to device")
