"""Test and benchmark scaffolding around the paged-KV library (not part of it).

workloads     seeded synthetic inputs: shapes, contexts, block tables, slots
device_cache  device pools of a workload filled through the library's own append
probe         streaming-read and copy yardstick kernels (``libpkvprobe.so``)
build_probe   builds ``libpkvprobe.so`` from ``csrc/pkv_probe.hip``

Only tests, the benchmark and the smoke check import this package; the library
package never does.
"""
