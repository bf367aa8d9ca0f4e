"""Seeded synthetic inputs shared by the tests, the bench and the smoke check."""
from .synth import (Layer, Workload, WORKLOAD_NAMES, make_workload, layer_inputs, features, weights,
                    sphere_shell, indoor_scene, lidar_frame, coarsen, batched_lidar, random_grid, permuted)
