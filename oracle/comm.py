"""Per-GPU forward communication volume of ring vs Ulysses attention.

Test infrastructure only (see the package docstring).  Design input for how
the path would shard across GPUs; no kernel depends on it.

[CP vs Ulysses], section "推导 / 关键公式": per GPU and layer, in elements,
ring attention receives cp - 1 KV blocks of 2 (s/cp) h_kv elements each, and
Ulysses all-to-alls Q, K, V and O, sending (cp-1)/cp of the local data.
h and h_kv are the hidden sizes (heads x head dim) of the queries and of the
KV; the bytes per element are 2 for bf16.
"""


def ring_elements(s, h_kv, cp):
    return 2 * s * h_kv * (cp - 1) / cp


def ulysses_elements(s, h, h_kv, cp):
    return (s / cp) * (2 * h + 2 * h_kv) * (cp - 1) / cp


def mib(elements, bytes_per_element=2):
    return elements * bytes_per_element / 2**20
