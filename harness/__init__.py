"""Device-side harness of the synthetic workloads: turns a seeded `synth` workload into the device state of one
step (caches holding each request's history, the step's new Q/K/V rows, buffers for outputs and partial results)
and drives the package's step pipeline over it, for the GPU tests, the benchmark and the smoke check.

Harness, not product: the package `paged_kv_attention_varlen_amd` knows nothing of workloads; this module only
marshals a workload's requests, pools and values into the package's calls. Position-to-slot arithmetic is the
library's (cb_slot_mapping, cb_build_metadata)."""
from .device_step import (build_step, fill_history, new_rows, pipeline_for, scheduler_for, sched_pools,  # noqa: F401
                          upload_new_rows)
