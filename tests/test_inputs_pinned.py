"""The bench's synthetic inputs are reproducible from their seeds: the
arrays bench.host_inputs generates for the short workloads (the ones whose
inputs a bench record's inputs_sha256 lists) hash to these pinned values, so
a record's hashes identify the exact inputs on any machine. A change to the
generator or to a workload's seeds shows up here first."""
import pytest

import bench
from fp4_quant_amd import inputs

PINNED = {
    "decode": [{"x": "f29ef7567e660e6c306a2b0c72986698ae03651a5d6c5cb30522fc1307f5e860",
                "gamma": "eb69165da262f55803700e0bc8c7e567a3796de595239cab768a91015c091ed5",
                "residual": "a7ada784d296c210a981c839f4f0dda6ad6c9b238cfc9b5530e6f29232bc8f6e"}],
    "prefill512": [{"x": "a6b48ab39dbf7049228c983294e0f03c0721fa618a2ec5dc0c7e0f93df047a5e",
                    "gamma": "eb69165da262f55803700e0bc8c7e567a3796de595239cab768a91015c091ed5",
                    "residual": "1ee0b630608e5761a14bca1387e747c273d423b1a564147a31e8331d58111673"}],
    "mla": [{"x": "b6afb206681d750caa4a383ed1aa121cb7f25b986fbc2f149f6a4d9959723e0a",
             "gamma": "3951edabf288c5eb84b2d3e783b558681861b06d7b31f9f7b3ab01b0b6976ef0"},
            {"x": "23623d47b9b0d711f09755e7fd999e40a7137b10022c6d0b2b0054a73e653408",
             "gamma": "f0e85ee7b865194021a9964a3d01add1446acfb8da56a7a06f7f690bebd3454c"}],
}


@pytest.mark.parametrize("name", sorted(PINNED))
def test_workload_inputs_hash_to_the_pinned_values(name):
    specs = bench.SPECS[name][0]
    got = [{k: inputs.sha256(v) for k, v in p.items() if hasattr(v, "dtype")} for p in bench.host_inputs(specs)]
    assert got == PINNED[name]
