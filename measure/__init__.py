"""Measurement probes for bench.py: plain moves of the engine's rows, one direction
per launch with nothing else in it (libprobes.so), next to copy-engine transfers of the
same bytes, so that the engine's host-link launch and gather can be set against the
plain form and the alternatives. Not part of the engine, and nothing in the engine
loads it."""
