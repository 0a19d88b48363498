"""Write tests/golden/perf_baseline.json from a `bench.py --all --json-out FILE` result.

The baseline is the last recorded run of every decode workload (its layered decode-call
time, the bench's roofline timing) on an MI355X; tests/test_zy_perf_smoke.py checks a
new run against it.  Usage: python tests/golden/perf_baseline.py FILE
"""
import json
import sys
from pathlib import Path


def main(path: str) -> None:
    d = json.loads(Path(path).read_text())
    us = {c["workload"]: round(float(c["decode_us_layered"]), 2) for c in d["configs"]}
    for o in d.get("others", []):
        us[o["workload"]] = round(float(o["decode_ms_layered"]) * 1e3, 2)
    out = {
        "source": "bench.py --all: layered decode-call mean (cold per-layer cache copies), MI355X",
        "decode_us_layered": us,
    }
    dst = Path(__file__).with_name("perf_baseline.json")
    dst.write_text(json.dumps(out, indent=1) + "\n")
    print(f"wrote {dst}: {us}")


if __name__ == "__main__":
    main(sys.argv[1])
