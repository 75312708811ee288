"""fp64 CPU oracle of Looped Latent Attention decode (test infrastructure).

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may
import this package; the product package never does."""
